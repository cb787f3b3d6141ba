/*
 * moe_mi355x.h -- C ABI of the sparse Mixture-of-Experts feed-forward layer
 * for AMD Instinct MI355X (gfx950).
 *
 * The layer is the block-sparse MoE of PhiMoE and its shared-expert
 * variants:
 *   - router: a bias-free linear layer from hidden size to the number of
 *     experts ("深入解析 Transformers 中的 PhiMoE" page, section 6, call chain
 *     of PhimoeSparseMoeBlock / PhimoeTopKRouter);
 *   - top-k experts per token with softmax weights over the selected
 *     experts (same page, section 6, sparsemixer at inference: greedy top-1,
 *     mask it, take the next, softmax the selected weights);
 *   - no token is ever dropped and no capacity padding is applied (same
 *     page, section 2, item 4);
 *   - experts are packed: gate_up_proj [E, 2I, H] (gate rows first, then up
 *     rows) and down_proj [E, H, I]; each expert computes
 *     down(silu(gate x) * up x) (same page, section 2, item 3);
 *   - tokens are sorted by expert id and grouped so that one grouped GEMM
 *     serves all experts ("Transformer中的混合专家架构详解" page, experts
 *     backends section, grouped_mm; weight-loading section: kernels need the
 *     experts packed in one contiguous tensor);
 *   - optional always-on shared expert added to the routed output
 *     (GraniteMoeSWA page, decoder-layer section: moe output + shared_mlp;
 *     Instella page, FarSkipMoE: routed + shared, routed scaling factor).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller; the
 *     library never allocates or frees memory on the call path and keeps no
 *     mutable global state (calls on different streams may overlap as long
 *     as their buffers do not). The one exception is moe_forward_noalloc:
 *     its per-GPU scratch array, and that array's address, looked up once
 *     per device (thread-safe) and then only read.
 *   - Tensors are dense, row-major, with the shapes stated; base pointers
 *     must be 16-byte aligned; H, I and shared_I must be multiples of 8.
 *   - Every argument check runs before any HIP call; a rejected call has
 *     enqueued nothing. Work is enqueued asynchronously on opts->stream and
 *     no host synchronisation happens; device faults surface at the caller's
 *     next synchronisation.
 *   - Error details of the last failing call on the calling thread are
 *     available from moe_last_error().
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = -1, /* bad shape, k, dtype, null pointer, aliasing  */
    MOE_ERR_UNSUPPORTED = -2, /* valid request outside what this build serves */
    MOE_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required   */
    MOE_ERR_ALIGNMENT = -4,   /* a pointer is not 16-byte aligned             */
    MOE_ERR_HIP = -5          /* a HIP launch or runtime call failed          */
} moe_status;

typedef enum moe_dtype {
    MOE_BF16 = 0, /* bf16 hidden, router, expert weights and output; fp32 accumulation */
    MOE_F32 = 1   /* fp32 everywhere                                                */
} moe_dtype;

/* How router logits become expert scores (opts->score_func). */
typedef enum moe_score_func {
    MOE_SCORE_SOFTMAX = 0, /* weights: softmax over the selected logits          */
    MOE_SCORE_SIGMOID = 1, /* scores sigmoid(logit); weights: the selected       */
                           /* scores divided by their sum                         */
    MOE_SCORE_SPARSEMIXER = 2 /* PhiMoE's sparsemixer at inference (see below)   */
} moe_score_func;

/* Storage of the routed experts' weights (gate_up, down). */
typedef enum moe_weight_format {
    MOE_WEIGHTS_NATIVE = 0,  /* same dtype as the activations (opts->dtype)          */
    MOE_WEIGHTS_FP8_E4M3 = 1, /* one byte per weight, OCP FP8 E4M3, plus one fp32   */
                             /* scale per weight row: w = e4m3(q) * scale (see      */
                             /* moe_quantize_fp8_rows); bf16 activations only        */
    MOE_WEIGHTS_MXFP4 = 2    /* OCP MX FP4: two E2M1 weights per byte and one E8M0 */
                             /* scale byte per 32 weights of a row (see            */
                             /* moe_quantize_mxfp4_rows); bf16 activations only     */
} moe_weight_format;

/* Storage order of the routed experts' bf16 weights (opts->weight_layout). */
typedef enum moe_weight_layout {
    MOE_LAYOUT_ROWS = 0,       /* gate_up [E, 2I, H], down [E, H, I]: nn.Linear rows */
    MOE_LAYOUT_TILE_BLOCKS = 1 /* the blocks moe_pack_tile_blocks writes            */
} moe_weight_layout;

/* which matrix moe_pack_tile_blocks / moe_tile_blocks_bytes describe */
#define MOE_PACK_GATE_UP 0
#define MOE_PACK_DOWN 1

/* opts->flags bits: choose the expert-GEMM schedule (default: by shape). */
#define MOE_FLAG_FORCE_TILED 0x1u  /* large-M tiles (prefill schedule)          */
#define MOE_FLAG_FORCE_SKINNY 0x2u /* weight-streaming tiles (decode schedule)  */

typedef struct moe_opts {
    uint32_t struct_size;     /* = sizeof(moe_opts); set by moe_opts_init            */
    int32_t dtype;            /* moe_dtype of hidden, router_w, gate_up, down, out,  */
                              /* shared_gate_up and shared_down                      */
    float routed_scale;       /* multiplies the routed weights only (default 1.0)   */
    uint32_t flags;           /* MOE_FLAG_* bits, default 0                          */
    const float *router_bias; /* [E] fp32 added to every logit row, or NULL          */
    const void *shared_gate_up; /* [2*shared_I, H] (gate rows then up rows) or NULL  */
    const void *shared_down;  /* [H, shared_I] or NULL                               */
    int64_t shared_I;         /* intermediate size of the shared expert; 0 = none    */
    /* Optional outputs (NULL = not written). */
    float *router_logits;     /* [T, E] fp32 logits, bias included                   */
    int32_t *topk_ids;        /* [T, k] selected experts, slot 0 = largest logit     */
    float *topk_weights;      /* [T, k] renormalised weights times routed_scale      */
    int32_t *expert_counts;   /* [E] assignments per expert                          */
    int32_t *expert_offsets;  /* [E+1] exclusive prefix sum of expert_counts         */
    int32_t *perm;            /* [T*k] sorted position -> flat assignment t*k+j      */
    int32_t *inv_perm;        /* [T*k] flat assignment -> sorted position            */
    /* Scratch memory, at least moe_workspace_bytes(...) bytes, 256-byte aligned. */
    void *workspace;
    size_t workspace_bytes;
    void *stream;             /* hipStream_t to enqueue on; NULL = default stream    */
    /* Optional stage timing: MOE_NUM_STAGE_EVENTS caller-created hipEvent_t
     * handles (or NULL). Event 0 is recorded on the stream before the first
     * kernel and event i+1 after stage i (see MOE_STAGE_*), so the time of
     * stage i is the elapsed time between events i and i+1. Stages that do
     * not run (no shared expert) take zero time. NULL entries are skipped. */
    void *const *stage_events;
    /* Routed expert weights stored as FP8 (moe_weight_format; default native).
     * With MOE_WEIGHTS_FP8_E4M3, gate_up is bytes [E, 2I, H] and down bytes
     * [E, H, I], each row scaled by gate_up_scale [E, 2I] / down_scale [E, H]
     * (fp32); H and I must be multiples of 16. This is the storage that
     * halves the bytes a decode step streams (MoEs in Transformers page,
     * section on why MoEs are fast: decode speed ~ bandwidth / bytes of the
     * active weights; per-expert quantisation once experts are packed). The
     * shared expert stays in opts->dtype. These weights run on the
     * weight-streaming kernels only: MOE_FLAG_FORCE_TILED is rejected, and so
     * are batches with T*k > 32*E (more than about 32 rows per expert, where
     * an expert's weights would be streamed once per 32 of its rows), with
     * MOE_ERR_UNSUPPORTED; the same holds for MOE_WEIGHTS_MXFP4. */
    int32_t weight_format;
    const float *gate_up_scale;
    const float *down_scale;
    /* Router statistics for the load-balancing auxiliary loss ("深入解析
     * Transformers 中的 PhiMoE" page, section 6: the Switch Transformer
     * load-balancing loss over the router logits, times router_aux_loss_coef
     * = 0.001, padding tokens excluded). Computed when any output below is
     * non-NULL, over the tokens with stats_mask[t] != 0 (all tokens when
     * stats_mask is NULL); n = number of such tokens:
     *   router_prob_mean[e] = (1/n) sum_t softmax(logits[t, :])[e]
     *                         (softmax over all E experts, bias included),
     *   expert_load[e]      = (1/n) #{(t, j): topk_ids[t, j] = e},
     *   aux_loss[0]         = E * sum_e expert_load[e] * router_prob_mean[e]
     *                         (the caller multiplies by its coefficient);
     * all zero when n = 0. Routing itself ignores stats_mask. */
    const int32_t *stats_mask; /* [T] or NULL                                   */
    float *router_prob_mean;   /* [E] or NULL                                   */
    float *expert_load;        /* [E] or NULL                                   */
    float *aux_loss;           /* [1] or NULL                                   */
    /* Scoring variants. The Instella page names its top-k method "noaux_tc"
     * on a DeepSeek-V3 base: sigmoid expert scores, a load-balancing bias
     * that steers selection only, and group-limited selection. The pages do
     * not spell these out; this follows DeepSeek-V3's published router.
     * Defaults (all zero) give the PhiMoE softmax router above.
     *
     * score_func = MOE_SCORE_SIGMOID: the score of expert e is
     * s = 1 / (1 + exp(-c)), c = the logit clamped to [-80, 80] (fmin/fmax:
     * a NaN logit becomes -80), in fp32 with
     * exp built from correctly rounded IEEE operations only, so it is the
     * same bit for bit on any conforming machine:
     *   n = rint(x * fl(1/ln2)); r = fma(-n, A, x); r = fma(-n, B, r) with
     *   A = 0.693145751953125 and B = fl(ln2 - A); p = Horner evaluation in
     *   fma of the Taylor polynomial sum_{j=0..8} fl(1/j!) r^j;
     *   exp(x) = ldexp(p, n)
     * (fl = round to nearest fp32). Selection ranks experts by
     * key = score + selection_bias[e] (score = the logit for softmax; the
     * ranking rule as above), while the weights use the unbiased scores of
     * the selected experts: softmax over the selected logits, or the
     * selected sigmoid scores divided by their sum, times routed_scale.
     *
     * n_group > 1: the E experts form n_group equal groups of consecutive
     * experts; a group's score is the fp32 sum, best first, of its best two
     * keys (its one key when E == n_group); the topk_group best groups (ties
     * to the lower group) are kept and the k experts are chosen among them.
     * Requires E % n_group == 0, 1 <= topk_group <= n_group and
     * k <= topk_group * E / n_group; otherwise MOE_ERR_INVALID_ARG.
     * selection_bias values must be finite.
     *
     * score_func = MOE_SCORE_SPARSEMIXER (PhiMoE page, section 6, the
     * sparsemixer router at inference; the threshold is the config's
     * router_jitter_noise): experts are chosen greedily by logit as for
     * softmax, and round j's weight is a softmax of its own. With m the
     * logit of the expert chosen in round j and R the experts not chosen in
     * earlier rounds, the round keeps the experts e of R with
     * NOT ((m - l[e]) / max(|l[e]|, m) > 2 * jitter_eps) (fp32 subtraction,
     * correctly rounded fp32 division, so a 0/0 keeps the expert), and
     * w_j = routed_scale / sum over the kept e of exp(l[e] - m). The weights
     * need not sum to routed_scale. No selection_bias or groups with it. */
    int32_t score_func;           /* moe_score_func                            */
    const float *selection_bias;  /* [E] fp32 added to selection keys, or NULL */
    int32_t n_group;              /* 0 or 1: no grouping                        */
    int32_t topk_group;
    float jitter_eps;             /* sparsemixer threshold; moe_opts_init sets */
                                  /* 0.01 (PhiMoE's router_jitter_noise)       */
    /* MOE_WEIGHTS_MXFP4: gate_up holds [E, 2I, H/2] bytes and down [E, H, I/2]
     * (codes of elements 2i and 2i+1 in the low and high nibble of byte i),
     * with E8M0 block scales gate_up_block_scale [E, 2I, H/32] and
     * down_block_scale [E, H, I/32] (byte arrays, any alignment; rows of
     * scales that start 4-byte aligned, K % 128 == 0 and a 4-byte aligned
     * array, are read 16 bytes at a time); H and I multiples of 32;
     * weight-streaming kernels only (MOE_FLAG_FORCE_TILED is rejected). */
    const uint8_t *gate_up_block_scale;
    const uint8_t *down_block_scale;
    /* MOE_LAYOUT_TILE_BLOCKS: gate_up and down hold the routed experts' bf16
     * weights as moe_pack_tile_blocks wrote them (bytes as
     * moe_tile_blocks_bytes gives). Every batch then runs on the large-M
     * tiled kernels, whose weight copies each read 1 KB contiguous instead of
     * 16 rows x 64 bytes ("Transformer中的混合专家架构详解" page, experts
     * backends: grouped_mm over packed expert weights; the packing here is a
     * storage order of the same weights). bf16, MOE_WEIGHTS_NATIVE only;
     * MOE_FLAG_FORCE_SKINNY is rejected; the shared expert keeps
     * MOE_LAYOUT_ROWS. Results are bit for bit those of MOE_LAYOUT_ROWS on the
     * tiled schedule (MOE_FLAG_FORCE_TILED). */
    int32_t weight_layout;
} moe_opts;

/* Stages of moe_forward, in launch order. */
enum {
    MOE_STAGE_ROUTER = 0,        /* router logits, top-k, weights, block histogram */
    MOE_STAGE_SCAN = 1,          /* expert counts, offsets, tile list              */
    MOE_STAGE_PERMUTE = 2,       /* stable expert-major permutation                */
    MOE_STAGE_GATE_UP = 3,       /* routed gate_up GEMM with fused silu(gate)*up   */
    MOE_STAGE_DOWN = 4,          /* routed down GEMM, weighted slot scatter        */
    MOE_STAGE_SHARED_GATE_UP = 5,
    MOE_STAGE_SHARED_DOWN = 6,
    MOE_STAGE_COMBINE = 7,       /* ordered slot sum (+ shared), output rounding   */
    MOE_NUM_STAGES = 8,
    MOE_NUM_STAGE_EVENTS = 9
};

/* Fills *opts with defaults: dtype MOE_BF16, routed_scale 1, everything else 0. */
void moe_opts_init(moe_opts *opts);

/*
 * Bytes of workspace moe_forward needs for these sizes and options (only
 * dtype, shared_I and flags of opts are read; opts may be NULL for the
 * defaults). Returns a negative moe_status when the sizes are invalid.
 * Pure host arithmetic: no HIP call.
 */
int64_t moe_workspace_bytes(int64_t T, int64_t H, int64_t I, int64_t E, int32_t k,
                            const moe_opts *opts);

/*
 * out[T, H] = sum over the k experts selected for each token of
 *             w[t, j] * down_e(silu(gate_e x_t) * up_e x_t)
 *             (+ shared expert output when opts->shared_I > 0).
 *
 * hidden   [T, H]       token activations
 * router_w [E, H]       router weight (nn.Linear layout [out, in])
 * gate_up  [E, 2I, H]   rows [0, I) gate projection, rows [I, 2I) up projection
 * down     [E, H, I]    down projection (nn.Linear layout [out, in])
 * out      [T, H]       written in full; must not overlap any input
 *
 * The workspace must not overlap any input; out, the workspace and the
 * optional outputs must not overlap each other (MOE_ERR_INVALID_ARG).
 * The number of compute units of the current device is queried on every
 * call (it sizes the persistent launches); nothing is cached between calls.
 *
 * Sizes: T >= 0 (T = 0 is a successful no-op), 1 <= k <= E <= 256, H, I >= 8
 * and multiples of 8, T*k < 2^31; one expert (2*I*H, 2*shared_I*H) and one
 * activation tensor (T*H, T*k*I, T*shared_I) below 2^31 elements, H, I and
 * shared_I at most 2^24 (else MOE_ERR_UNSUPPORTED).
 *
 * Routing is reproducible bit for bit. The logit of expert e is an fp32 sum
 * of products hidden[t,i]*router_w[e,i] taken in this order: 64 partial sums
 * P[0..63], element i = 512c + 8L + v (v = 0..7) fused-multiply-added into
 * P[L] with c ascending, then v ascending; then for d = 32, 16, 8, 4, 2, 1
 * every P[L] becomes P[L] + P[L xor d]; the logit is P[0] + router_bias[e].
 * Experts rank by logit, ties to the lower index, a NaN key below every
 * number (so every token gets k valid experts whatever its inputs; its
 * weights and outputs are then NaN); slot j of a token holds its j-th
 * ranked expert. Weights are exp(l_j - l_0) / sum_i exp(l_i - l_0)
 * over the selected experts, times routed_scale. Assignments are grouped by
 * expert, ascending t*k+j inside each group.
 *
 * Returns MOE_OK or a negative moe_status; on error nothing was enqueued
 * unless the status is MOE_ERR_HIP (a launch failed part-way).
 */
int moe_forward(const void *hidden, const void *router_w, const void *gate_up, const void *down,
                int64_t T, int64_t H, int64_t I, int64_t E, int32_t k, const moe_opts *opts,
                void *out);

/* Scratch bytes that moe_forward_noalloc holds on each GPU it runs on. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

/*
 * moe_forward without a caller workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops and
 * harnesses that forbid hipMalloc. Same arguments, results and checks as
 * moe_forward, except:
 *   - opts->workspace must be NULL and opts->workspace_bytes 0
 *     (MOE_ERR_INVALID_ARG otherwise); the layer's scratch lives in a device
 *     array of MOE_NOALLOC_SCRATCH_BYTES inside the library, one per GPU,
 *     held until the process ends;
 *   - sizes whose workspace (moe_workspace_bytes) exceeds that array are
 *     rejected with MOE_ERR_UNSUPPORTED (the PhiMoE decode step, T = 32,
 *     H = 4096, I = 6400, E = 16, k = 2, needs about 2 MB, a 256-token
 *     batch of the same layer about 91 MB; large prefill calls need more:
 *     use moe_forward for those);
 *   - no call allocates or frees memory; the first call on a device looks up
 *     the array's address on that device once (hipGetSymbolAddress, with
 *     that device current) and keeps it for later calls;
 *   - every call on one GPU uses the same array, which keeps the last call's
 *     contents (every call writes what it reads first, nothing needs
 *     clearing). Calls that overlap in time on one GPU (other streams, or
 *     other host threads without ordering) race on it; calls ordered on one
 *     stream do not.
 */
int moe_forward_noalloc(const void *hidden, const void *router_w, const void *gate_up, const void *down,
                        int64_t T, int64_t H, int64_t I, int64_t E, int32_t k, const moe_opts *opts,
                        void *out);

/*
 * Per-row FP8 quantisation of a bf16 matrix w [rows, cols] (for instance the
 * packed gate_up viewed as [E*2I, H], or down as [E*H, I]):
 *   a = max_i |w[r, i]|,  scale[r] = a / 448 (fp32 division; 1 when a = 0),
 *   q[r, i] = the OCP FP8 E4M3 value nearest to w[r, i] / scale[r] (fp32
 *             division), ties to the even code, saturating at +-448; zero
 *             is stored as 0x00.
 * E4M3: sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent
 * field 0 holds the subnormals m * 2^-9; 0x7F / 0xFF are NaN (never
 * produced). 448 is the largest finite magnitude.
 * q [rows, cols] bytes and scale [rows] fp32 are device outputs; cols >= 16
 * and a multiple of 16; w and q 16-byte aligned. Asynchronous on stream
 * (hipStream_t, NULL = default). Returns MOE_OK or a negative moe_status
 * (argument checks run before any HIP call).
 */
int moe_quantize_fp8_rows(const void *w, int64_t rows, int64_t cols, void *q, float *scale, void *stream);

/*
 * The routed experts' bf16 weights in tile blocks (MOE_LAYOUT_TILE_BLOCKS),
 * written once from the nn.Linear layout; every block is one 32-column
 * k-stage of one 256-row weight block of the tiled kernels, so each stage of
 * a tile streams one contiguous 16 KB run. Zero where a row or column lies
 * past the matrix.
 *   MOE_PACK_GATE_UP, w = gate_up [E, 2I, H]: out [E][NB = ceil(I/128)]
 *     [NK = ceil(H/32)][256][32]; in block (e, nb, kt), row r < 128 holds gate
 *     row nb*128 + r of expert e and row 128 + r holds up row
 *     I + nb*128 + r, columns kt*32 .. kt*32 + 31;
 *   MOE_PACK_DOWN, w = down [E, H, I]: out [E][NB = ceil(H/256)]
 *     [NK = ceil(I/32)][256][32]; row r of block (e, nb, kt) holds row
 *     nb*256 + r of expert e, columns kt*32 .. kt*32 + 31.
 * moe_tile_blocks_bytes returns E * NB * NK * 16384 (or a negative
 * moe_status for bad arguments: which, E >= 1, H and I positive multiples
 * of 8, one expert's blocks below 2^31 bytes). moe_pack_tile_blocks writes
 * them: w and out device buffers, 16-byte aligned, not overlapping;
 * asynchronous on stream (hipStream_t, NULL = default); argument errors are
 * returned before any HIP call.
 */
int64_t moe_tile_blocks_bytes(int32_t which, int64_t E, int64_t I, int64_t H);
int moe_pack_tile_blocks(int32_t which, const void *w, int64_t E, int64_t I, int64_t H, void *out, void *stream);

/*
 * MXFP4 quantisation (OCP Microscaling Formats v1.0, MXFP4) of a bf16 matrix
 * w [rows, cols], in blocks of 32 consecutive elements of a row:
 *   a = the block's largest magnitude; x = floor(log2 a) - 2 (2 = the largest
 *   E2M1 exponent), clamped to [-127, 127], -127 when a < 2^-126;
 *   scale byte = x + 127 (E8M0: the block's factor is 2^x);
 *   each code = the E2M1 value nearest to w / 2^x, ties to the even code,
 *   magnitudes past 6 saturating to 6, sign bit = w's sign bit.
 * E2M1 code: bit 3 sign, bits 2..1 exponent e (bias 1), bit 0 mantissa m;
 * e = 0 gives m * 0.5, otherwise 2^(e-1) * (1 + m/2): 0, 0.5, 1, 1.5, 2, 3,
 * 4, 6. The weight is code value * 2^x (exactly a bf16 value).
 * q [rows, cols/2] bytes (element 2i in the low nibble of byte i, 2i+1 in the
 * high nibble) and scale [rows, cols/32] bytes are device outputs; cols a
 * positive multiple of 32; w 16-byte aligned. Asynchronous on stream
 * (hipStream_t, NULL = default). Returns MOE_OK or a negative moe_status
 * (argument errors before any HIP call).
 */
int moe_quantize_mxfp4_rows(const void *w, int64_t rows, int64_t cols, void *q, void *scale, void *stream);

/* Message describing the last failing call on this thread ("" if none). */
const char *moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
